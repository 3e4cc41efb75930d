"""GPU check of moe_decode_layer_noalloc, the variant of moe_decode_layer whose workspace is a device array
held by the library (for callers that cannot allocate): through the C ABI, its outputs equal
moe_decode_layer's on a fresh caller workspace bit for bit, on consecutive calls with a smaller shape after a
larger one (and the larger again), and a shape beyond the array's size is rejected before anything runs."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from bit_quantized_expert_int8_amd import moeq4 as q  # noqa: E402
import gpu_helpers as H  # noqa: E402


def _pools(cfg, dev, shape):
    rp = q.pool(dev.pool, dev.pool.shape[1], shape.n_experts, shape.d, shape.F, shape.sb_dtype)
    sp = q.pool(dev.shared, dev.shared.shape[1], 1, shape.d, shape.S, shape.sb_dtype)
    return rp, sp


def _outputs(cfg, x):
    return (torch.full((cfg.k,), -7, dtype=torch.int32, device="cuda"),
            torch.full((cfg.k,), -1.0, dtype=torch.float32, device="cuda"),
            torch.full((cfg.n_experts,), -1.0, dtype=torch.float32, device="cuda"),
            torch.zeros_like(x), torch.zeros_like(x))


def _both(cfg, dev, shape, tok, status):
    """(no-alloc outputs, caller-workspace outputs) for one token: ids, weights, logits, u, out."""
    x = H.token_batch(cfg, [tok])[0]
    xdt = q.MOE_BF16 if cfg.x_bf16 else q.MOE_F32
    gamma = dev.gamma if cfg.rms_norm else None
    rp, sp = _pools(cfg, dev, shape)
    a = _outputs(cfg, x)
    q.moe_decode_layer_noalloc(x, xdt, gamma, 1e-6, int(cfg.rms_norm), dev.router_w, dev.router_s, cfg.n_experts,
                               cfg.k, None, rp, None, sp, shape.act, a[0], a[1], a[2], a[3], a[4], status)
    b = _outputs(cfg, x)
    wsb = q.moe_decode_layer_workspace_bytes(cfg.d, cfg.n_experts, cfg.k, cfg.F, cfg.S)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    q.moe_decode_layer(x, xdt, gamma, 1e-6, int(cfg.rms_norm), dev.router_w, dev.router_s, cfg.n_experts, cfg.k,
                       None, rp, None, sp, shape.act, b[0], b[1], b[2], b[4], ws, wsb, u=b[3])
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    return a, b


def test_noalloc_equals_caller_workspace_on_consecutive_shapes():
    big, small = synth.STACK, synth.TINY
    dev_big, dev_small = H.device_layer(big, 0), H.device_layer(small, 0)
    shape_big, shape_small = H.shape_of(big), H.shape_of(small)
    assert q.moe_decode_layer_workspace_bytes(big.d, big.n_experts, big.k, big.F, big.S) <= \
        q.MOE_DECODE_LAYER_NOALLOC_MAX_BYTES
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    calls = [(big, dev_big, shape_big, 3), (small, dev_small, shape_small, 5), (big, dev_big, shape_big, 9),
             (big, dev_big, shape_big, 9), (small, dev_small, shape_small, 6)]
    for n, (cfg, dev, shape, tok) in enumerate(calls):
        print(f"no-alloc call {n}: d={cfg.d} E={cfg.n_experts} k={cfg.k} token {tok}", flush=True)
        a, b = _both(cfg, dev, shape, tok, status)
        for name, ta, tb in zip(("ids", "weights", "logits", "u", "out"), a, b):
            assert torch.equal(ta, tb), f"call {n}: {name} differs from the caller-workspace call"
        assert int(status.item()) == 0, f"call {n}: a bounded wait ran out"
        assert sorted(a[0].cpu().tolist()) == sorted(set(a[0].cpu().tolist())) and min(a[0].cpu().tolist()) >= 0


def test_noalloc_rejects_a_shape_beyond_the_array():
    # d = 4096, 256 experts, top-32, F = 1024, shared 4096 needs about 1.4 MB: refused on the host, nothing runs
    cfg = synth.TINY
    dev = H.device_layer(cfg, 0)
    d, E, k, F, S = 4096, 256, 32, 1024, 4096
    need = q.moe_decode_layer_workspace_bytes(d, E, k, F, S)
    assert need > q.MOE_DECODE_LAYER_NOALLOC_MAX_BYTES
    rb, srb = q.moe_record_bytes(d, F, q.MOE_BF16), q.moe_record_bytes(d, S, q.MOE_BF16)
    rp = q.pool(dev.pool, rb, E, d, F, q.MOE_BF16)       # never read: the call is refused first
    sp = q.pool(dev.shared, srb, 1, d, S, q.MOE_BF16)
    x = torch.zeros(d, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(x)
    st = q.raw("moe_decode_layer_noalloc")(x.data_ptr(), q.MOE_BF16, None, 1e-6, 0, dev.router_w.data_ptr(),
                                           dev.router_s.data_ptr(), E, k, None, q.ctypes.byref(rp), None,
                                           q.ctypes.byref(sp), q.MOE_ACT_GELU_TANH, None, None, None, None,
                                           out.data_ptr(), None, None)
    assert st == q.MOE_ERR_UNSUPPORTED
    assert "more than" in q.moe_last_error()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
