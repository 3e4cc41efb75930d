"""C-ABI library checks that need no GPU: exported symbols, record layout, host-side argument validation,
and the LFU cache policy run in host-only mode against the oracle's policy simulation."""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT
import synth
from oracle import moe

q = pytest.importorskip("bit_quantized_expert_int8_amd.moeq4", reason="libmoeq4.so not built")


def _header_functions():
    src = open(os.path.join(ROOT, "include", "moeq4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(q.LIB_PATH)
    names = _header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/moeq4.h but not exported"
    assert set(names) == set(q.EXPORTED)


@pytest.mark.parametrize("compiler,flags", [("gcc", ["-x", "c", "-std=c99"]), ("g++", ["-x", "c++", "-std=c++17"])])
def test_header_compiles_alone(compiler, flags, tmp_path):
    """include/moeq4.h is a self-contained C header: it compiles on its own as C99 and as C++17, warning-free."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    src = tmp_path / "use_header.c"
    src.write_text('#include "moeq4.h"\nint main(void) { return 0; }\n')
    r = subprocess.run([compiler, *flags, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.parametrize("d,F,sb", [(256, 128, 0), (2816, 704, 1), (2816, 2816, 1), (64, 64, 0), (4096, 1536, 1)])
def test_record_layout_matches_oracle(d, F, sb):
    lay = moe.record_layout(d, F, sb == 1)
    assert q.moe_record_bytes(d, F, sb) == lay.total
    assert q.moe_record_layout(d, F, sb) == (lay.gate_up_q, lay.gate_up_sb, lay.down_q, lay.down_sb)


def test_record_bytes_rejects_bad_shapes():
    assert q.moe_record_bytes(100, 64, 1) == 0
    assert q.moe_record_bytes(64, 0, 1) == 0
    assert q.moe_record_bytes(64, 64, 7) == 0


def _status(name, *args):
    return q.raw(name)(*args)


def test_host_validation_errors():
    assert _status("q4_quantize", None, 4, 64, 1, 16, 16, None) == q.MOE_ERR_INVALID_ARG
    assert _status("q4_quantize", 16, 4, 60, 1, 16, 16, None) == q.MOE_ERR_INVALID_ARG
    assert "multiple of 64" in q.moe_last_error()
    # q4_gemv: K not a multiple of 64, K too large, N = 0, T = 0, NULL codes, misaligned x, bad dtype
    g = lambda x, T, codes, N, K, sbt=1: _status("q4_gemv", x, 0, T, codes, 256, sbt, N, K, 256, None)
    assert g(256, 1, 256, 16, 96) == q.MOE_ERR_INVALID_ARG and "multiple of 64" in q.moe_last_error()
    assert g(256, 1, 256, 16, 8256) == q.MOE_ERR_INVALID_ARG
    assert g(256, 1, 256, 0, 64) == q.MOE_ERR_INVALID_ARG
    assert g(256, 0, 256, 16, 64) == q.MOE_ERR_INVALID_ARG
    assert g(256, 1, None, 16, 64) == q.MOE_ERR_INVALID_ARG and "NULL" in q.moe_last_error()
    assert g(256 + 4, 1, 256, 16, 64) == q.MOE_ERR_INVALID_ARG and "aligned" in q.moe_last_error()
    assert g(256, 1, 256, 16, 64, sbt=7) == q.MOE_ERR_INVALID_ARG
    assert _status("moe_rmsnorm", 16, 1, 16, ctypes.c_float(1e-6), 0, 64, 16, 1, None) == q.MOE_ERR_INVALID_ARG
    # k > E, E too large, d not a multiple of 16
    args = lambda T, d, E, k, ws: (256, 1, T, d, 256, 256, E, k, None, 256, 256, None, 256, ws, None)
    assert _status("moe_router_topk", *args(1, 64, 8, 9, 1 << 20)) == q.MOE_ERR_UNSUPPORTED
    assert _status("moe_router_topk", *args(1, 64, 2048, 8, 1 << 20)) == q.MOE_ERR_UNSUPPORTED
    assert _status("moe_router_topk", *args(1, 60, 8, 2, 1 << 20)) == q.MOE_ERR_UNSUPPORTED
    assert _status("moe_router_topk", *args(1, 64, 8, 2, 16)) == q.MOE_ERR_INVALID_ARG      # workspace too small
    assert q.moe_router_workspace_bytes(1, 128) == 256 + 512
    # one ticket counter per token, 256 bytes apart, then the logits [T][E] fp32
    assert q.moe_router_workspace_bytes(32, 128) == 32 * 256 + 32 * 128 * 4
    # q4_expert_gemv: misaligned pool, mismatched d, k too large
    bad = q.pool(256 + 16, 61440, 8, 256, 128, 0)
    good = q.pool(256, 61440, 8, 256, 128, 0)
    sh = q.pool(1 << 20, 61440, 1, 512, 128, 0)
    st = q.raw("q4_expert_gemv")
    assert st(ctypes.byref(bad), 256, 2, None, 256, 0, 1, 0, 256, None, 256, 1 << 20, None) == q.MOE_ERR_INVALID_ARG
    assert st(ctypes.byref(good), 256, 2, ctypes.byref(sh), 256, 0, 1, 0, 256, 256, 256, 1 << 20, None) == q.MOE_ERR_INVALID_ARG
    assert st(ctypes.byref(good), 256, 33, None, 256, 0, 1, 0, 256, None, 256, 1 << 20, None) == q.MOE_ERR_UNSUPPORTED
    assert st(ctypes.byref(good), 256, 2, None, 256, 0, 1, 0, 256, None, 256, 16, None) == q.MOE_ERR_INVALID_ARG
    assert q.q4_expert_gemv_workspace_bytes(good, 2, None, 1) == 1024
    assert _status("moe_combine", None, None, None, None, 0, 1, 2, 64, 256, 0, None) == q.MOE_ERR_INVALID_ARG
    # fused gemv + combine: hidden activations (1024) + y_routed (2*256*4) + one counter per 16 rows (16*4 -> 256)
    assert q.q4_expert_gemv_combine_workspace_bytes(good, 2, None, 1) == 1024 + 2048 + 256
    fc = q.raw("q4_expert_gemv_combine")
    fargs = lambda w, out, ws: (ctypes.byref(good), 256, 2, None, 256, 1, 1, 0, w, None, 1, out, 1, 256, ws, None)
    assert fc(*fargs(256, None, 1 << 20)) == q.MOE_ERR_INVALID_ARG                       # out NULL
    assert fc(*fargs(None, 256, 1 << 20)) == q.MOE_ERR_INVALID_ARG                       # weights NULL with k > 0
    assert fc(*fargs(256, 256, 3328 - 256)) == q.MOE_ERR_INVALID_ARG                     # no room for the counters
    assert "workspace" in q.moe_last_error()
    # batched (T = 3): hidden activations 3*2*128*4 = 3072, then the grouping tables: the group and chunk
    # counts (256), min(T*k, n_records + 1) = 6 groups of 16 bytes (-> 256), at most 6 + T*k/16 = 6 chunks
    # of 16 pairs (-> 256), T*k pair indices (-> 256) and room for the work descriptors of the two grouped
    # launches (2 x 4096 x 16 bytes); then the rows staged for the matrix cores, the larger of the tokens
    # (3 x 256 fp16 = 1536, 3 x 4 groups x 8 bytes -> 256, 3 row scales -> 256) and the hidden vectors
    # (6 x 128 fp16 = 1536, 6 x 2 x 8 -> 256, 6 -> 256)
    assert q.q4_expert_gemv_workspace_bytes(good, 2, None, 3) == 3072 + 256 + 256 + 256 + 256 + 2 * 4096 * 16 + 2048
    assert q.moe_group_pairs_max_groups(32, 8, 128) == 129 and q.moe_group_pairs_max_groups(1, 8, 128) == 8
    gp = q.raw("moe_group_pairs")
    assert gp(256, 4, 2, 5000, 256, 256, 256, None) == q.MOE_ERR_UNSUPPORTED          # pool too large to group
    assert gp(256, 4, 2, 8, 256, 256 + 4, 256, None) == q.MOE_ERR_INVALID_ARG         # groups not 16-byte aligned
    assert gp(256, 0, 2, 8, 256, 256, 256, None) == q.MOE_ERR_INVALID_ARG             # T = 0
    big = q.pool(256, 61440, 5000, 256, 128, 0)
    assert st(ctypes.byref(big), 256, 2, None, 256, 0, 2, 0, 256, None, 256, 1 << 24, None) == q.MOE_ERR_UNSUPPORTED
    # a batch whose staged rows (T*k rows of the longest row, fp16) would pass 2 GiB: 65535 * 32 * 1024 * 2
    wide = q.pool(256, q.moe_record_bytes(1024, 512, 0), 8, 1024, 512, 0)
    assert st(ctypes.byref(wide), 256, 32, None, 256, 0, 65535, 0, 256, None, 256, 1 << 40, None) == q.MOE_ERR_UNSUPPORTED
    assert "2 GiB" in q.moe_last_error()
    # stacked layers: 1..32 layers, out must not alias x
    stk = q.raw("moe_decode_stack")
    one = q.stack_layers([{"router_w_dev": 256, "router_scale_dev": 256, "routed_base_dev": 256}])
    assert stk(one, 0, 256, 1, ctypes.c_float(1e-6), 1, 8, 2, ctypes.byref(good), None, 0, 512, 256, 1 << 24,
               None) == q.MOE_ERR_UNSUPPORTED
    assert stk(one, 1, 256, 1, ctypes.c_float(1e-6), 1, 8, 2, ctypes.byref(good), None, 0, 256, 256, 1 << 24,
               None) == q.MOE_ERR_INVALID_ARG
    assert q.moe_decode_stack_workspace_bytes(33, 256, 8, 2, 128, 128) == 0
    assert q.moe_decode_stack_workspace_bytes(3, 256, 8, 2, 128, 128) == 3 * q.moe_decode_layer_workspace_bytes(
        256, 8, 2, 128, 128)
    # fused norm + router: gamma and u are required, eps must be >= 0
    nr = q.raw("moe_norm_router_topk")
    nargs = lambda g, eps, u: (256, 1, g, ctypes.c_float(eps), 1, 64, 256, 256, 8, 2, None, 256, 256, None, u, 256,
                               1 << 20, None)
    assert nr(*nargs(None, 1e-6, 256)) == q.MOE_ERR_INVALID_ARG
    assert nr(*nargs(256, 1e-6, None)) == q.MOE_ERR_INVALID_ARG
    assert nr(*nargs(256, -1.0, 256)) == q.MOE_ERR_INVALID_ARG
    with pytest.raises(q.MoeError):
        q.q4_quantize(None, 4, 64, 1, 16, 16)


# ---------------------------------------------------------------------------------------------------
# LFU cache in host-only mode
# ---------------------------------------------------------------------------------------------------

class HostCache:
    def __init__(self, n_layers, n_experts, n_slots, rb=64, seed=0):
        rng = np.random.default_rng(seed)
        self.rb = rb
        self.host = [rng.integers(0, 256, size=(n_experts, rb), dtype=np.uint8) for _ in range(n_layers)]
        self.slots = [np.zeros((n_slots, rb), dtype=np.uint8) for _ in range(n_layers)]
        self.n_slots = n_slots
        self.h = q.moe_expert_cache_create(n_layers, n_experts, n_slots, rb, [a.ctypes.data for a in self.host],
                                           [a.ctypes.data for a in self.slots], q.MOE_CACHE_HOST_ONLY)
        self.out = np.zeros(32, dtype=np.int32)

    def stage(self, layer, ids):
        q.expert_cache_stage(self.h, layer, ids, self.out.ctypes.data)
        return self.out[:len(ids)].tolist()

    def held(self, layer):
        return q.moe_expert_cache_slots(self.h, layer, self.n_slots)

    def close(self):
        q.moe_expert_cache_destroy(self.h)


def test_cache_hand_worked_trace(golden_dir):
    rows = [r for r in open(os.path.join(golden_dir, "lfu_trace_small.txt")) if r.strip() and not r.startswith("#")]
    c = HostCache(1, 10, int(rows[0].split()[1]))
    total_hits = 0
    for row in rows[1:]:
        _, ids, slots, hits, held = [x.split() for x in row.split("|")]
        assert c.stage(0, [int(v) for v in ids]) == [int(v) for v in slots]
        assert c.held(0) == [int(v) for v in held]
        total_hits += int(hits[0])
    h, m, b = q.moe_expert_cache_stats(c.h, 0)
    assert (h, m, b) == (total_hits, 14 - total_hits, (14 - total_hits) * c.rb)
    c.close()


def test_cache_matches_oracle_on_zipf_trace():
    L, T, k, E = 3, 400, 8, 128
    tr = synth.zipf_trace(21, T, L, k, E, 1.1)
    slots, hits = moe.lfu_simulate(tr, 16)
    c = HostCache(L, E, 16)
    for t in range(T):
        for l in range(L):
            assert c.stage(l, tr[t, l]) == slots[t, l].tolist()
            for i, e in enumerate(tr[t, l]):      # slot bytes == host record bytes
                assert np.array_equal(c.slots[l][slots[t, l, i]], c.host[l][e])
    for l in range(L):
        h, m, _ = q.moe_expert_cache_stats(c.h, l)
        assert h == hits[:, l].sum() and h + m == T * k
    c.close()


def test_cache_errors_and_transactional_failure():
    c = HostCache(2, 32, 4)
    with pytest.raises(q.MoeError) as ei:
        c.stage(0, [1, 1])
    assert ei.value.status == q.MOE_ERR_CACHE
    with pytest.raises(q.MoeError) as ei:
        c.stage(0, [1, 2, 3, 4, 5])
    assert ei.value.status == q.MOE_ERR_CACHE
    with pytest.raises(q.MoeError) as ei:
        c.stage(0, [40])
    assert ei.value.status == q.MOE_ERR_OUT_OF_RANGE
    with pytest.raises(q.MoeError) as ei:
        c.stage(2, [1])
    assert ei.value.status == q.MOE_ERR_OUT_OF_RANGE
    c.stage(0, [1, 2])
    c.stage(0, [3, 4])            # all four slots full
    before = c.held(0)
    stats = q.moe_expert_cache_stats(c.h, 0)
    # the second copy of the next call fails: nothing is committed, the slot that got the first copy is emptied
    q.moe_expert_cache_inject_copy_failure(c.h, 1)
    with pytest.raises(q.MoeError) as ei:
        c.stage(0, [5, 6, 1])
    assert ei.value.status == q.MOE_ERR_HIP
    after = c.held(0)
    assert q.moe_expert_cache_stats(c.h, 0) == stats
    changed = [s for s in range(4) if after[s] != before[s]]
    assert len(changed) == 1 and after[changed[0]] == -1
    # the failure was one-shot: the same request now succeeds and the policy continues from the kept state
    slots = c.stage(0, [5, 6, 1])
    assert sorted(c.held(0)[s] for s in slots) == [1, 5, 6]
    c.close()
