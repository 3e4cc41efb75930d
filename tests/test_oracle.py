"""Pins of the CPU oracle against things other than itself: hand-worked fixtures, closed forms,
special cases that reduce to textbook or library routines, and brute force on tiny inputs."""
import math
import os

import numpy as np
import pytest
import scipy.special

import synth
from oracle import moe
from oracle import inputs as oin


def _read_fixture(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ---------------------------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------------------------

def test_f64_round_to_bf16_matches_bit_rounding_of_f32():
    # an independent route: the generator's bit-trick RNE on fp32 inputs (exactly representable in f64)
    x = synth.normals_f32(synth.stream_seed(9, 0, 0), 0, 20000, 3.0)
    via_bits = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(moe.f64_round_to_bf16(x.astype(np.float64)), via_bits)
    assert np.array_equal(moe.f32_round_to_bf16(x).astype(np.float64), via_bits)


def test_f64_round_to_bf16_ties():
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 3 * 2 ** -8 + 1 + 2 ** -30, 0.0, -2.0], dtype=np.float64)
    assert list(moe.f64_round_to_bf16(x)) == [1.0, 1 + 2 ** -6, 1 + 2 ** -6, 0.0, -2.0]


# ---------------------------------------------------------------------------------------------
# packing, quantizer, dequantizer, record layout
# ---------------------------------------------------------------------------------------------

def test_nibble_order_fixture(golden_dir):
    rows = _read_fixture(golden_dir, "nibble_order.txt")
    codes = np.array([int(v) for v in rows[0].split(":")[1].split()], dtype=np.uint8)[None, :]
    words = np.array([int(v, 16) for v in rows[1].split(":")[1].split()], dtype=np.uint32)[None, :]
    assert np.array_equal(moe.pack_codes(codes), words)
    assert np.array_equal(moe.unpack_codes(words), codes)


def test_quantize_hand_fixture(golden_dir):
    rows = dict(r.split(":", 1) for r in _read_fixture(golden_dir, "quantize_hand.txt"))
    a = (0.5 * (np.arange(64) % 16) - 2.0).astype(np.float32)
    b = np.full(64, 3.0, dtype=np.float32)
    cvals = [float(v) for v in rows["groupC_values"].split()]
    c = np.full(64, float(rows["groupC_fill_value"]), dtype=np.float32)
    c[:len(cvals)] = cvals
    w = np.concatenate([a, b, c])[None, :]
    for sb_bf16 in (False, True):
        q, s, bias = moe.quantize_affine_q4(w, sb_bf16)
        assert list(s[0]) == [0.5, 0.0, 1.0] and list(bias[0]) == [-2.0, 3.0, 0.0]
        assert np.array_equal(q[0, :64], np.arange(64) % 16)
        assert np.all(q[0, 64:128] == 0)
        expect_c = [int(v) for v in rows["groupC_codes"].split()]
        assert list(q[0, 128:128 + len(expect_c)]) == expect_c
        assert np.all(q[0, 128 + len(expect_c):] == int(rows["groupC_fill_code"]))
        deq = moe.dequantize(q, s, bias)
        assert np.array_equal(deq[0, :128], np.concatenate([a, b]).astype(np.float64))


@pytest.mark.parametrize("sb_bf16", [False, True])
def test_quantize_round_trip_bound(sb_bf16):
    w = synth.weight_f32(5, 0, 2, 0, 96, 512)
    q, s, b = moe.quantize_affine_q4(w, sb_bf16)
    assert q.min() >= 0 and q.max() <= 15
    deq = moe.dequantize(q, s, b)
    u = 2.0 ** -9 if sb_bf16 else 2.0 ** -24
    g = w.reshape(96, 8, 64).astype(np.float64)
    mn = g.min(axis=2)
    bound = (s.astype(np.float64) / 2 * (1 + 2.0 ** -18) + u * (np.abs(mn) + 16 * s)) + 1e-12
    err = np.abs(deq.reshape(96, 8, 64) - g).max(axis=2)
    assert np.all(err <= bound)
    # the bound is tight to within the half-step: most groups use it
    assert np.median(err / (s / 2)) > 0.9


def test_quantize_fp32_minimum_exact_and_constant_group():
    w = synth.weight_f32(5, 1, 2, 0, 16, 128)
    w[3, 64:] = -0.25
    q, s, b = moe.quantize_affine_q4(w, False)
    deq = moe.dequantize(q, s, b)
    g = w.reshape(16, 2, 64)
    r, gi = np.unravel_index(np.arange(32), (16, 2))
    for rr, gg in zip(r, gi):
        j = int(np.argmin(g[rr, gg]))
        assert deq[rr, gg * 64 + j] == float(g[rr, gg, j])
    assert s[3, 1] == 0 and np.all(deq[3, 64:] == -0.25)


def test_dequantize_row_sum_closed_form():
    # sum_c w_hat[r][c] = sum_g (s_g * sum_{c in g} q_c + 64 * b_g): a route through code sums only
    w = synth.weight_f32(5, 2, 2, 0, 24, 256)
    q, s, b = moe.quantize_affine_q4(w, True)
    qs = q.reshape(24, 4, 64).astype(np.float64).sum(axis=2)
    closed = (s.astype(np.float64) * qs + 64 * b.astype(np.float64)).sum(axis=1)
    assert np.allclose(moe.dequantize(q, s, b).sum(axis=1), closed, rtol=0, atol=1e-12)


def test_record_layout_sizes():
    # tiny config (fp32 scale/bias): 32768 + 8192 + 16384 + 4096 bytes
    lay = moe.record_layout(256, 128, False)
    assert (lay.gate_up_q, lay.gate_up_sb, lay.down_q, lay.down_sb, lay.total) == (0, 32768, 40960, 57344, 61440)
    # d=2816, F=704, bf16 scale/bias: 1982464 + 247808 + 991232 + 123904 bytes
    lay = moe.record_layout(2816, 704, True)
    assert (lay.gate_up_sb, lay.down_q, lay.down_sb, lay.total) == (1982464, 2230272, 3221504, 3345408)
    # shared expert of width 2816: 2x the gate/up rows, 4x the down columns
    assert moe.record_layout(2816, 2816, True).total == 13381632


def test_record_encode_decode_round_trip():
    d, F = 128, 64
    wgu = synth.weight_f32(5, 3, 2, 0, 2 * F, d)
    wd = synth.weight_f32(5, 3, 3, 0, d, F)
    for sb_bf16 in (False, True):
        rec = moe.encode_record(wgu, wd, sb_bf16)
        assert rec.size == moe.record_layout(d, F, sb_bf16).total
        dec = moe.decode_record(rec, d, F, sb_bf16)
        q, s, b = moe.quantize_affine_q4(wgu, sb_bf16)
        assert np.array_equal(dec.gate_up_codes, q) and np.array_equal(dec.gate_up_scale, s)
        assert np.array_equal(dec.gate_up_bias, b)
        q, s, b = moe.quantize_affine_q4(wd, sb_bf16)
        assert np.array_equal(dec.down_codes, q) and np.array_equal(dec.down_bias, b)


# ---------------------------------------------------------------------------------------------
# expert FFN on exactly representable weights (quantization lossless) vs raw weights, loop by loop
# ---------------------------------------------------------------------------------------------

def _grid_weights(rng, rows, cols):
    # every group holds codes 0..15 at scale 1/8 and a per-group offset: lossless under the quantizer
    q = rng.integers(0, 16, size=(rows, cols))
    q[:, ::64] = 0
    q[:, 1::64] = 15
    off = rng.integers(-8, 8, size=(rows, cols // 64)).repeat(64, axis=1) / 8.0
    return (q / 8.0 + off).astype(np.float32)


@pytest.mark.parametrize("act", [moe.ACT_GELU_TANH, moe.ACT_SILU])
def test_expert_ffn_lossless_record_equals_loops(act):
    rng = np.random.default_rng(0)
    d, F = 128, 64
    wgu = _grid_weights(rng, 2 * F, d)
    wd = _grid_weights(rng, d, F)
    u = rng.standard_normal(d)
    rec = moe.encode_record(wgu, wd, True)
    y = moe.expert_ffn(moe.decode_record(rec, d, F, True), u, act)
    f = (lambda z: 0.5 * z * (1 + math.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))) \
        if act == moe.ACT_GELU_TANH else (lambda z: z * scipy.special.expit(z))
    h = []
    for j in range(F):
        g = sum(float(wgu[j, c]) * u[c] for c in range(d))
        v = sum(float(wgu[F + j, c]) * u[c] for c in range(d))
        h.append(f(g) * v)
    expect = [sum(float(wd[r, j]) * h[j] for j in range(F)) for r in range(d)]
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# activations
# ---------------------------------------------------------------------------------------------

def test_gelu_tanh_vs_exact_gelu():
    z = np.linspace(-8, 8, 20001)
    exact = 0.5 * z * (1 + scipy.special.erf(z / math.sqrt(2)))
    err = np.abs(moe.gelu_tanh(z) - exact)
    assert err.max() < 5e-4          # the tanh form tracks the erf form to a few 1e-4
    assert moe.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(moe.gelu_tanh(z) - moe.gelu_tanh(-z), z, atol=1e-12)


def test_silu_vs_library_sigmoid():
    z = np.linspace(-30, 30, 6001)
    assert np.allclose(moe.silu(z), z * scipy.special.expit(z), rtol=1e-13, atol=1e-15)
    assert np.allclose(moe.silu(z) - moe.silu(-z), z, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------------------------

def test_router_logits_special_cases():
    E, d = 6, 64
    s = np.array([0.5, 0.25, 2.0, 1.0, 0.125, 4.0], dtype=np.float32)
    w = np.zeros((E, d), dtype=np.int8)
    for e in range(E):
        w[e, e] = 127                # expert e reads only input e
    u = np.zeros(d)
    u[2] = 1.0
    assert list(moe.router_logits(w, s, u)) == [0, 0, 2.0 * 127, 0, 0, 0]
    w2 = np.tile(np.arange(-3, 3, dtype=np.int8)[:, None], (1, d))   # row e constant e-3
    u2 = np.full(d, 0.5)
    assert np.allclose(moe.router_logits(w2, s, u2), s * (np.arange(E) - 3) * 0.5 * d, rtol=0, atol=0)


def test_topk_fixture(golden_dir):
    for row in _read_fixture(golden_dir, "topk_hand.txt"):
        lg, k, ids = row.split("|")
        got = moe.select_topk(np.array([float(v) for v in lg.split()]), int(k))
        assert list(got) == [int(v) for v in ids.split()]


def test_topk_brute_force_small():
    rng = np.random.default_rng(1)
    for _ in range(300):
        n = int(rng.integers(1, 9))
        lg = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties
        k = int(rng.integers(1, n + 1))
        brute = sorted(range(n), key=lambda e: (-lg[e], e))[:k]
        assert list(moe.select_topk(lg, k)) == brute


def test_gate_weights_closed_forms():
    assert np.allclose(moe.gate_weights(np.array([1.0, 1.0 + math.log(3)]), [1, 0]), [0.75, 0.25])
    assert moe.gate_weights(np.array([5.0, -2.0]), [1]) == pytest.approx([1.0])
    lg = np.random.default_rng(2).standard_normal(128) * 3
    ids = moe.select_topk(lg, 8)
    w = moe.gate_weights(lg, ids)
    assert abs(w.sum() - 1.0) < 1e-15 and np.all(np.diff(w) <= 0)
    # softmax over all experts renormalised over the kept ones (library softmax)
    p = scipy.special.softmax(lg)[ids]
    assert np.allclose(w, p / p.sum(), rtol=1e-13)


# ---------------------------------------------------------------------------------------------
# whole layer: dense brute force, k = E, x = 0
# ---------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny_layer():
    return oin.oracle_layer(synth.TINY, 0, cache_experts=8)


def test_tiny_layer_sparse_equals_dense_brute_force(tiny_layer):
    cfg = synth.TINY
    for t in range(3):
        u = oin.token_input(cfg, t)
        res = moe.moe_layer(tiny_layer, u, cfg.k)
        dense = moe.dense_moe_layer(tiny_layer, u, cfg.k, cfg.n_experts)
        assert np.allclose(res.out, dense, rtol=0, atol=1e-12 * np.abs(dense).max())
        assert abs(res.weights.sum() - 1) < 1e-12


def test_tiny_layer_k_equals_E_is_softmax_moe(tiny_layer):
    cfg = synth.TINY
    u = oin.token_input(cfg, 5)
    res = moe.moe_layer(tiny_layer, u, cfg.n_experts)
    p = scipy.special.softmax(res.logits)
    ys = [moe.expert_ffn(tiny_layer.decoded(e), u, moe.ACT_GELU_TANH) for e in range(cfg.n_experts)]
    expect = sum(p[e] * ys[e] for e in range(cfg.n_experts)) + res.y_shared
    assert np.allclose(res.out, expect, rtol=0, atol=1e-12 * np.abs(expect).max())
    assert sorted(res.ids.tolist()) == list(range(cfg.n_experts))


def test_tiny_layer_zero_input(tiny_layer):
    cfg = synth.TINY
    res = moe.moe_layer(tiny_layer, np.zeros(cfg.d), cfg.k, residual=np.full(cfg.d, 0.5))
    assert list(res.ids) == list(range(cfg.k))
    assert np.allclose(res.weights, 1.0 / cfg.k)
    assert np.all(res.out == 0.5)


def test_tiny_layer_forced_ids(tiny_layer):
    cfg = synth.TINY
    u = oin.token_input(cfg, 1)
    res = moe.moe_layer(tiny_layer, u, cfg.k, forced_ids=[6, 3])
    assert list(res.ids) == [6, 3]
    lg = res.logits
    assert res.weights[0] == pytest.approx(1 / (1 + math.exp(lg[3] - lg[6])))


# ---------------------------------------------------------------------------------------------
# RMSNorm and the stacked step
# ---------------------------------------------------------------------------------------------

def test_rms_norm_closed_forms():
    d = 64
    assert np.allclose(moe.rms_norm(np.full(d, -3.0), np.ones(d), 0.0), -1.0)
    x = np.random.default_rng(3).standard_normal(d)
    u = moe.rms_norm(x, np.ones(d), 0.0)
    assert abs(np.mean(u * u) - 1) < 1e-12
    assert np.allclose(moe.rms_norm(7.5 * x, np.ones(d), 0.0), u, rtol=1e-13)
    g = np.linspace(0.5, 1.5, d)
    assert np.allclose(moe.rms_norm(x, g, 0.0), u * g, rtol=1e-13)


def test_stack_step_rounding_points(tiny_layer):
    cfg = synth.TINY
    x = moe.f64_round_to_bf16(oin.token_input(cfg, 2))
    u, res, xn = moe.stack_layer_step(tiny_layer, x, cfg.k)
    assert np.array_equal(moe.f64_round_to_bf16(u), u)
    assert np.array_equal(moe.f64_round_to_bf16(xn), xn)
    assert np.allclose(xn, res.out, rtol=2 ** -8, atol=0)
    assert np.allclose(res.out - x, moe.combine(res.y_routed, res.weights, res.y_shared), atol=1e-12)


# ---------------------------------------------------------------------------------------------
# LFU expert cache
# ---------------------------------------------------------------------------------------------

def test_lfu_hand_worked_trace(golden_dir):
    rows = _read_fixture(golden_dir, "lfu_trace_small.txt")
    n_slots = int(rows[0].split()[1])
    sim = moe.LfuCacheSim(n_slots)
    for row in rows[1:]:
        _, ids, slots, hits, held = [c.split() for c in row.split("|")]
        st = sim.step([int(v) for v in ids])
        assert st.slots == [int(v) for v in slots]
        assert st.hits == int(hits[0])
        assert sim.expert == [int(v) for v in held]


def test_lfu_invariants_on_zipf_trace():
    tr = synth.zipf_trace(11, 300, 3, 8, 128, 1.1)
    slots, hits = moe.lfu_simulate(tr, 16)
    assert slots.min() >= 0 and slots.max() < 16
    for t in range(tr.shape[0]):
        for l in range(tr.shape[1]):
            assert len(set(slots[t, l].tolist())) == 8
    assert 0 < hits.sum() < tr.shape[0] * tr.shape[1] * 8


def test_lfu_few_distinct_experts_miss_once():
    rng = np.random.default_rng(4)
    pool = rng.choice(128, 16, replace=False)
    tr = np.array([[rng.choice(pool, 8, replace=False)] for _ in range(100)])
    slots, hits = moe.lfu_simulate(tr, 16)
    misses = tr.size - hits.sum()
    assert misses == len(np.unique(tr))


def test_lfu_relabel_invariant():
    tr = synth.zipf_trace(12, 100, 1, 8, 128, 1.1)
    perm = np.random.default_rng(5).permutation(128)
    s1, h1 = moe.lfu_simulate(tr, 16)
    s2, h2 = moe.lfu_simulate(perm[tr], 16)
    assert np.array_equal(s1, s2) and np.array_equal(h1, h2)


# ---------------------------------------------------------------------------------------------
# grouping of (token, slot) pairs by expert
# ---------------------------------------------------------------------------------------------

def test_group_pairs_hand_fixture(golden_dir):
    rows = [r.split() for r in _read_fixture(golden_dir, "group_pairs_hand.txt")]
    ids = np.array([[int(v) for v in r[1:]] for r in rows if r[0] == "ids"])
    perm = [int(v) for r in rows if r[0] == "perm" for v in r[1:]]
    groups = [tuple(int(v) for v in r[1:]) for r in rows if r[0] == "group"]
    g, p = moe.group_pairs(ids, 4)
    assert p.tolist() == perm
    assert g == groups


def test_group_pairs_brute_force_and_invariants():
    """Against a bucket-by-bucket scan of the pairs (a different construction), plus the invariants:
    perm is a permutation, buckets ascend along perm, pairs ascend within a bucket, counts = histogram."""
    rng = np.random.default_rng(5)
    for T, k, n in ((1, 8, 128), (5, 3, 8), (32, 8, 128), (7, 4, 3)):
        ids = rng.integers(-2, n + 3, size=(T, k))
        g, p = moe.group_pairs(ids, n)
        flat = ids.reshape(-1)
        bucket_of = [e if 0 <= e < n else n for e in flat.tolist()]
        scan, ref_groups = [], []
        for b in range(n + 1):
            members = [q for q in range(T * k) if bucket_of[q] == b]
            if members:
                ref_groups.append((b, len(scan), len(members)))
            scan += members
        assert p.tolist() == scan and g == ref_groups
        assert sorted(p.tolist()) == list(range(T * k))
        bs = [bucket_of[q] for q in p.tolist()]
        assert bs == sorted(bs)
        assert np.array_equal(np.bincount(bs, minlength=n + 1), np.bincount(bucket_of, minlength=n + 1))


# ---------------------------------------------------------------------------------------------
# the C expert FFN (oracle/fast.py) against the numpy definition, and the many-token evaluator
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("sb_bf16", [False, True])
def test_c_quantizer_equals_numpy_bit_for_bit(sb_bf16):
    from oracle import fast
    w = synth.normals_f32(synth.stream_seed(7, 1, synth.TAG_GATE_UP, 3), 0, 96 * 256, 0.02).reshape(96, 256)
    w[3, :64] = 0.25                                     # constant group: scale 0, codes 0
    w[4, 64:128] = (0.5 * (np.arange(64) % 16) - 2.0)    # exact grid with ties at half steps
    w[5, 128:192] = np.linspace(-1, 1, 64) ** 3
    c1, s1, b1 = fast.quantize_q4(w, sb_bf16)
    c2, s2, b2 = moe.quantize_affine_q4(w, sb_bf16)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(b1.view(np.uint32), b2.view(np.uint32))


@pytest.mark.parametrize("act", [moe.ACT_GELU_TANH, moe.ACT_SILU])
def test_c_expert_ffn_equals_numpy(act):
    from oracle import fast
    cfg = synth.TINY
    U = np.stack([oin.token_input(cfg, t) for t in range(5)] + [np.zeros(cfg.d)])
    for e in (0, 5):
        wgu, wd = oin.expert_weights(cfg, 0, e)
        ex = moe.decode_record(moe.encode_record(wgu, wd, cfg.sb_bf16), cfg.d, cfg.F, cfg.sb_bf16)
        y, h = fast.expert_ffn_rows(wgu, wd, cfg.sb_bf16, U, act, want_h=True)
        for t in range(len(U)):
            ref = moe.expert_ffn(ex, U[t], act)
            assert np.allclose(y[t], ref, rtol=0, atol=1e-12 * max(np.abs(ref).max(), 1e-300))
            assert np.allclose(h[t], moe.expert_hidden(ex, U[t], act), rtol=0, atol=1e-12 * np.abs(h[t]).max() + 1e-300)
        assert np.all(y[-1] == 0.0)                       # x = 0 -> y = 0 exactly


def test_c_expert_ffn_lossless_grid_equals_loops():
    # weights on the quantizer's grid, so the encoding is lossless: the C FFN must equal explicit loops over
    # the fp32 weights (a computation that never sees the encoder)
    from oracle import fast
    rng = np.random.default_rng(1)
    d, F = 128, 64
    wgu, wd = _grid_weights(rng, 2 * F, d), _grid_weights(rng, d, F)
    u = rng.standard_normal(d)
    y = fast.expert_ffn_rows(wgu, wd, True, u[None, :], moe.ACT_SILU)[0]
    h = []
    for j in range(F):
        g = sum(float(wgu[j, c]) * u[c] for c in range(d))
        v = sum(float(wgu[F + j, c]) * u[c] for c in range(d))
        h.append(g * scipy.special.expit(g) * v)
    expect = [sum(float(wd[r, j]) * h[j] for j in range(F)) for r in range(d)]
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_layer_tokens_equals_moe_layer_tiny(tiny_layer):
    from oracle import fast
    cfg = synth.TINY
    X = np.stack([oin.token_input(cfg, t) for t in range(6)])
    ids = np.stack([moe.select_topk(moe.router_logits(tiny_layer.router_w, tiny_layer.router_s, X[t]), cfg.k)
                    for t in range(6)])
    ids[2] = [7, 0]                                       # a forced selection in the middle
    res = fast.layer_tokens(cfg, 0, X, ids, threads=3)
    for t in range(6):
        ref = moe.moe_layer(tiny_layer, X[t], cfg.k, forced_ids=ids[t])
        assert np.array_equal(res[t].ids, ref.ids)
        assert np.allclose(res[t].weights, ref.weights, rtol=0, atol=1e-15)
        assert np.allclose(res[t].out, ref.out, rtol=0, atol=1e-12 * np.abs(ref.out).max())
        assert np.array_equal(res[t].x_next, res[t].out)  # fp32 configuration: no output rounding


def test_layer_tokens_equals_stack_step_full_size():
    """One token through one full-size stacked layer (d=2816, 128 experts top-8, shared 2816, RMSNorm +
    residual, bf16): the many-token evaluator equals moe.stack_layer_step (numpy) on the same routing."""
    from oracle import fast
    cfg = synth.STACK
    orc = oin.oracle_layer(cfg, 3, cache_experts=8)
    x = oin.token_input(cfg, 11)
    u, ref, x_next = moe.stack_layer_step(orc, x, cfg.k)
    res = fast.layer_tokens(cfg, 3, x[None, :], ref.ids[None, :])[0]
    assert np.array_equal(res.u, u)
    assert np.allclose(res.logits, ref.logits, rtol=0, atol=1e-12)
    assert np.allclose(res.out, ref.out, rtol=0, atol=1e-12 * np.abs(ref.out).max())
    assert np.array_equal(res.x_next, x_next)
